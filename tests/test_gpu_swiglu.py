"""GPU parity of sg_swiglu_gemm, sg_interleave_gate_up and sg_silu_mul against
the fp64 oracle (through the C ABI).

SwiGLU workload of the gated-MLP page ("Resumo Técnico: Sobreposição de Ativação
em Nível de Tile ...", Definição do Problema / Kernel-2): A [M x 896] ~ N(0,1),
W1, W2 [896 x 4864] ~ N(0, 0.02^2) column-interleaved into W_fused [896 x 9728],
M in {128, 512, 2048, 8192}."""
import numpy as np
import pytest

import oracle
from swiglu_gemm_amd import inputs
from helpers import split_count, assert_close, bits_equal, from_dev, to_dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import swiglu_gemm_amd as sg
    sg.lib()
    yield


def run_swiglu(A_bits, Wf_bits, M, N, K, dtype, sa=1.0, sw=1.0):
    import swiglu_gemm_amd as sg
    A = to_dev(A_bits, dtype)
    W = to_dev(Wf_bits, dtype)
    od = "f16" if dtype == "f16" else "bf16"
    Y = torch.full((M, N), float("nan"), device="cuda:0",
                   dtype=torch.float16 if od == "f16" else torch.bfloat16)
    print("swiglu %s M=%d N=%d K=%d" % (dtype, M, N, K), flush=True)
    sg.swiglu_gemm(A, W, Y, sa, sw)
    torch.cuda.synchronize()
    return from_dev(Y), sg.last_config()


def interleave_on_gpu(W1, W2, dtype):
    import swiglu_gemm_amd as sg
    return from_dev(sg.interleave_gate_up(to_dev(W1, dtype), to_dev(W2, dtype)))


@pytest.mark.parametrize("dtype,K,N", [("bf16", 5, 7), ("bf16", 896, 4864), ("f16", 3, 1),
                                       ("e4m3", 64, 130), ("f32", 17, 33)])
def test_interleave_bit_exact(dtype, K, N):
    gen = np.random.default_rng(3)
    st = inputs.STORAGE[dtype]
    if dtype == "f32":
        W1 = gen.standard_normal((K, N)).astype(np.float32)
        W2 = gen.standard_normal((K, N)).astype(np.float32)
    else:
        W1 = gen.integers(0, np.iinfo(st).max, size=(K, N)).astype(st)
        W2 = gen.integers(0, np.iinfo(st).max, size=(K, N)).astype(st)
    got = interleave_on_gpu(W1, W2, dtype)
    assert bits_equal(got, oracle.interleave(W1, W2))
    a, b = oracle.deinterleave(got)
    assert bits_equal(a, W1) and bits_equal(b, W2)


@pytest.mark.parametrize("M", [128, 512, 2048, 8192])
def test_swiglu_bf16_full(M):
    """Every output of the bf16 SwiGLU workload (K = 896, N = 4864) at each of its
    token counts, in the default launch configuration."""
    N, K = 4864, 896
    pb = inputs.swiglu_problem(4, M, N, K, "bf16")
    Wf = interleave_on_gpu(pb["W1"], pb["W2"], "bf16")
    y, cfg = run_swiglu(pb["A"], Wf, M, N, K, "bf16")
    ref = oracle.swiglu(M, N, K, pb["A"], Wf, "bf16")
    assert_close(oracle.decode(y, "bf16"), ref, "bf16", K, "swiglu bf16 M=%d %s" % (M, cfg),
                 report=True)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("shape", [(1, 1, 1), (7, 33, 40), (130, 100, 72), (300, 260, 200),
                                   (64, 512, 4096)])
def test_swiglu_ragged_shapes(dtype, shape):
    M, N, K = shape
    pb = inputs.swiglu_problem(44, M, N, K, dtype, w_std=0.1)
    Wf = oracle.interleave(pb["W1"], pb["W2"])
    y, cfg = run_swiglu(pb["A"], Wf, M, N, K, dtype)
    ref = oracle.swiglu(M, N, K, pb["A"], Wf, dtype)
    assert_close(oracle.decode(y, dtype), ref, dtype, K, "swiglu %s %s" % (shape, cfg))


@pytest.mark.parametrize("shape", [(96, 64, 64), (256, 512, 128), (70, 100, 2048)])
def test_swiglu_one_hot_bit_exact(shape):
    """W1, W2 select columns of A.  Gate sources are powers of two >= 32, where
    SiLU(g) rounds to g in fp32; up sources are integers in [-3, 3].  Then
    Y = g*u is exact in bf16, and a swapped gate/up or a shifted column shows."""
    M, N, K = shape
    gen = np.random.default_rng(K + N)
    half = K // 2
    A = np.zeros((M, K))
    A[:, :half] = 2.0 ** gen.integers(5, 9, size=(M, half)) * gen.choice([-1.0, 1.0], size=(M, half))
    A[:, :half] = np.abs(A[:, :half])      # SiLU(-g) is not -g: keep gates positive
    A[:, half:] = gen.integers(-3, 4, size=(M, K - half))
    pi1 = gen.integers(0, half, size=N)
    pi2 = half + gen.integers(0, K - half, size=N)
    W1 = np.zeros((K, N))
    W2 = np.zeros((K, N))
    W1[pi1, np.arange(N)] = 1.0
    W2[pi2, np.arange(N)] = 1.0
    Ab = inputs.to_storage(A, "bf16")
    Wf = oracle.interleave(inputs.to_storage(W1, "bf16"), inputs.to_storage(W2, "bf16"))
    y, cfg = run_swiglu(Ab, Wf, M, N, K, "bf16")
    expect = A[:, pi1] * A[:, pi2]
    assert np.array_equal(oracle.decode(y, "bf16"), expect), cfg


def test_swiglu_k_zero_writes_zero():
    import swiglu_gemm_amd as sg
    A = torch.zeros((4, 0), dtype=torch.bfloat16, device="cuda:0")
    W = torch.zeros((0, 10), dtype=torch.bfloat16, device="cuda:0")
    Y = torch.full((4, 5), 7.0, dtype=torch.bfloat16, device="cuda:0")
    # K == 0: the pointers may be anything non-NULL; pass a real allocation
    dummy = torch.zeros(8, dtype=torch.bfloat16, device="cuda:0")
    import ctypes
    st = sg.lib().sg_swiglu_gemm(ctypes.c_void_p(dummy.data_ptr()), ctypes.c_void_p(dummy.data_ptr()),
                                 ctypes.c_void_p(Y.data_ptr()), 4, 5, 0, 2, 1.0, 1.0, None)
    assert st == 0
    torch.cuda.synchronize()
    assert torch.all(Y == 0)
    del A, W


def test_swiglu_deterministic_and_split_k():
    M, N, K = 64, 512, 4096
    pb = inputs.swiglu_problem(45, M, N, K, "bf16")
    Wf = oracle.interleave(pb["W1"], pb["W2"])
    y1, cfg = run_swiglu(pb["A"], Wf, M, N, K, "bf16")
    y2, _ = run_swiglu(pb["A"], Wf, M, N, K, "bf16")
    assert bits_equal(y1, y2)
    assert split_count(cfg) > 1, cfg
    ref = oracle.swiglu(M, N, K, pb["A"], Wf, "bf16")
    assert_close(oracle.decode(y1, "bf16"), ref, "bf16", K, cfg)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_silu_mul(dtype):
    import swiglu_gemm_amd as sg
    gen = np.random.default_rng(8)
    for M, N in ((1, 1), (3, 13), (512, 4864)):
        G = inputs.to_storage(gen.standard_normal((M, N)) * 4, dtype)
        U = inputs.to_storage(gen.standard_normal((M, N)), dtype)
        Y = torch.empty((M, N), dtype=torch.float16 if dtype == "f16" else torch.bfloat16,
                        device="cuda:0")
        sg.silu_mul(to_dev(G, dtype), to_dev(U, dtype), Y)
        torch.cuda.synchronize()
        g = oracle.decode(G, dtype)
        u = oracle.decode(U, dtype)
        ref = np.array([oracle.silu(x) for x in g.ravel()]).reshape(M, N) * u
        assert_close(oracle.decode(from_dev(Y), dtype), ref, dtype, 1, "silu_mul")
