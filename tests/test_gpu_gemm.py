"""GPU parity of sg_gemm against the fp64 oracle (through the C ABI).

Covers: the worked 2x3x2 example bit-exactly in every dtype and transpose; fp32
256^3 with alpha/beta and the four transposes at 64x48x32; fp16 8192^3 (every
output) and multi-tile ragged fp16 shapes; bf16 NN/NT/TN/TT on 1000^3 and
4097x3001x2049 with padded leading dimensions (every output); identity/permutation products that
must be bit-exact; beta == 0 with NaN in C_old; K == 0 / alpha == 0 / empty
shapes; unaligned pointers and leading dimensions; split-K; determinism; and that
the ld padding of C is never written."""
import itertools
import json
import os

import numpy as np
import pytest

import oracle
from swiglu_gemm_amd import inputs
from helpers import split_count, TOL, assert_close, bits_equal, from_dev, out_dtype, to_dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TRANS = ["".join(t) for t in itertools.product("NT", "NT")]


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import swiglu_gemm_amd as sg
    sg.lib()
    yield


def run_gemm(p, ta, tb, M, N, K, alpha, beta, dtype):
    import swiglu_gemm_amd as sg
    A = to_dev(p["A"], dtype)
    B = to_dev(p["B"], dtype)
    C = to_dev(p["C"], out_dtype(dtype))
    print("gemm %s %s%s M=%d N=%d K=%d alpha=%g beta=%g" % (dtype, ta, tb, M, N, K, alpha, beta),
          flush=True)
    sg.gemm(A, B, C, alpha=alpha, beta=beta, transA=ta, transB=tb, M=M, N=N, K=K,
            lda=p["lda"], ldb=p["ldb"], ldc=p["ldc"],
            dtype={"f32": 0, "f16": 1, "bf16": 2, "e4m3": 3}[dtype])
    torch.cuda.synchronize()
    return from_dev(C), sg.last_config()


def check_full(p, ta, tb, M, N, K, alpha, beta, dtype, what="", report=False):
    cbits, cfg = run_gemm(p, ta, tb, M, N, K, alpha, beta, dtype)
    od = out_dtype(dtype)
    ref = oracle.gemm(ta, tb, M, N, K, alpha, p["A"], p["lda"], p["B"], p["ldb"], beta, p["C"],
                      p["ldc"], dtype, c_dtype=od)
    got = oracle.decode(cbits, od)
    assert_close(got[:, :N], ref[:, :N], od, K, "%s %s%s %s" % (what, ta, tb, cfg),
                 report=report)
    assert bits_equal(cbits[:, N:], p["C"][:, N:]), "ld padding of C was written"
    return cbits


# --------------------------------------------------------------------------
# worked example ("GEMM o Coração Matemático" §1): bit-exact in every dtype
# --------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("tr", TRANS)
def test_worked_example_bit_exact(dtype, tr, golden_dir):
    g = json.load(open(os.path.join(golden_dir, "worked_example_2x3x2.json")))
    ta, tb = tr
    A = np.array(g["A"], float)
    B = np.array(g["B"], float)
    As = inputs.to_storage(A.T if ta == "T" else A, dtype)
    Bs = inputs.to_storage(B.T if tb == "T" else B, dtype)
    for alpha, beta, cold, want in ((1.0, 0.0, np.full((2, 2), np.nan), g["AB"]),
                                    (g["alpha"], g["beta"], np.array(g["C_old"], float),
                                     g["C_alpha_beta"])):
        C = inputs.to_storage(cold, dtype)
        p = dict(A=As, B=Bs, C=C, lda=As.shape[1], ldb=Bs.shape[1], ldc=2)
        cbits, _ = run_gemm(p, ta, tb, 2, 2, 3, alpha, beta, dtype)
        assert np.array_equal(oracle.decode(cbits, dtype), np.array(want, float))


# --------------------------------------------------------------------------
# fp32: M=N=K=256, alpha=1.5, beta=0.5, U[-1,1]; four transposes at 64x48x32
# --------------------------------------------------------------------------

def test_f32_256_cube():
    p = inputs.gemm_problem(1, "N", "N", 256, 256, 256, "f32", "uniform")
    check_full(p, "N", "N", 256, 256, 256, 1.5, 0.5, "f32", "f32 256^3", report=True)


@pytest.mark.parametrize("tr", TRANS)
def test_f32_transposes_64x48x32(tr):
    p = inputs.gemm_problem(1, tr[0], tr[1], 64, 48, 32, "f32", "uniform")
    check_full(p, tr[0], tr[1], 64, 48, 32, 1.5, 0.5, "f32", "f32 64x48x32")


@pytest.mark.parametrize("tr", TRANS)
@pytest.mark.parametrize("shape,ld_mode,tile", [((3600, 3500, 129), "padded", 128),
                                                ((3599, 3601, 77), "tight", 128),
                                                ((1001, 1003, 517), "tight", 64)])
def test_f32_multi_tile(tr, shape, ld_mode, tile):
    """fp32 past one tile: 128 x 128 tiles (more than one round of them) and 64 x 64
    tiles, ragged edges and K tails, 16-byte loads (padded leading dimensions) and
    element loads (odd leading dimensions); every output against the oracle."""
    import swiglu_gemm_amd as sg
    M, N, K = shape
    p = inputs.gemm_problem(3, tr[0], tr[1], M, N, K, "f32", "uniform", ld_mode=ld_mode)
    check_full(p, tr[0], tr[1], M, N, K, 1.5, 0.5, "f32", "f32 %dx%dx%d" % shape)
    assert "gemm_f32 %dx%dx16" % (tile, tile) in sg.last_config(), sg.last_config()


# --------------------------------------------------------------------------
# fp16
# --------------------------------------------------------------------------

@pytest.mark.parametrize("tr", TRANS)
@pytest.mark.parametrize("shape", [(512, 512, 512), (700, 300, 520), (257, 1031, 129), (33, 17, 1000)])
def test_f16_multi_tile_ragged(tr, shape):
    M, N, K = shape
    p = inputs.gemm_problem(2, tr[0], tr[1], M, N, K, "f16", "normal", scale=1.0 / np.sqrt(K),
                            beta_zero=True)
    check_full(p, tr[0], tr[1], M, N, K, 1.0, 0.0, "f16", "f16 ragged")


def test_f16_8192_cube_full():
    """The square fp16 workload at full size, alpha=1, beta=0, C_old = NaN, in the
    configuration the benchmark times: every one of the 8192 x 8192 outputs against
    the oracle (about 25 s of oracle time on 16 host cores)."""
    M = N = K = 8192
    p = inputs.gemm_problem(2, "N", "N", M, N, K, "f16", "normal", scale=1.0 / np.sqrt(K),
                            beta_zero=True)
    cbits, cfg = run_gemm(p, "N", "N", M, N, K, 1.0, 0.0, "f16")
    got = oracle.decode(cbits, "f16")
    assert np.all(np.isfinite(got)), "NaN/Inf in C (C_old NaN must not leak at beta=0)"
    ref = oracle.gemm("N", "N", M, N, K, 1.0, p["A"], p["lda"], p["B"], p["ldb"], 0.0, p["C"],
                      p["ldc"], "f16")
    assert_close(got, ref, "f16", K, "f16 8192^3 NN " + cfg, report=True)


# --------------------------------------------------------------------------
# bf16 ragged shapes with padded ld, alpha=0.7, beta=0.3
# --------------------------------------------------------------------------

@pytest.mark.parametrize("tr", TRANS)
def test_bf16_1000_cube(tr):
    p = inputs.gemm_problem(3, tr[0], tr[1], 1000, 1000, 1000, "bf16", "normal", ld_mode="padded")
    assert p["lda"] == 1032 and p["ldb"] == 1032 and p["ldc"] == 1032
    check_full(p, tr[0], tr[1], 1000, 1000, 1000, 0.7, 0.3, "bf16", "bf16 1000^3", report=True)


@pytest.mark.parametrize("tr", TRANS)
def test_bf16_4097x3001x2049_full(tr):
    """Every output of the ragged bf16 workload (alpha=0.7, beta=0.3, leading
    dimensions padded to a multiple of 64 plus 8), and the padding of C untouched."""
    M, N, K = 4097, 3001, 2049
    p = inputs.gemm_problem(3, tr[0], tr[1], M, N, K, "bf16", "normal", ld_mode="padded")
    check_full(p, tr[0], tr[1], M, N, K, 0.7, 0.3, "bf16", "bf16 4097x3001x2049", report=True)


# --------------------------------------------------------------------------
# bit-exact layout: identity and permutation products
# --------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("tr", TRANS)
def test_identity_and_permutation_bit_exact(dtype, tr):
    ta, tb = tr
    M, K = 301, 267
    gen = np.random.default_rng(17)
    A = inputs.to_storage(gen.standard_normal((M, K)), dtype)     # op(A) values
    Avals = oracle.decode(A, dtype)
    perm = gen.permutation(K)
    P = np.zeros((K, K))
    P[np.arange(K), perm] = 1.0
    for Mat, expect in ((np.eye(K), Avals), (P, Avals[:, np.argsort(perm)])):
        As = A.T.copy() if ta == "T" else A
        Bv = Mat.T if tb == "T" else Mat
        lda = inputs.ld_padded(As.shape[1])
        ldb = inputs.ld_padded(Bv.shape[1])
        ldc = inputs.ld_padded(K)
        pA = inputs.padded(np.ascontiguousarray(As), lda, inputs.NAN_BITS[dtype])
        pB = inputs.padded(inputs.to_storage(Bv, dtype), ldb, inputs.NAN_BITS[dtype])
        nanC = np.full((M, K), np.nan)
        pC = inputs.padded(inputs.to_storage(nanC, dtype), ldc, inputs.SENTINEL[dtype])
        p = dict(A=pA, B=pB, C=pC, lda=lda, ldb=ldb, ldc=ldc)
        cbits, cfg = run_gemm(p, ta, tb, M, K, K, 1.0, 0.0, dtype)
        assert np.array_equal(oracle.decode(cbits[:, :K], dtype), expect), (dtype, tr, cfg)
        assert bits_equal(cbits[:, K:], pC[:, K:])


# --------------------------------------------------------------------------
# alpha / beta semantics and quick returns
# --------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_k_zero_and_alpha_zero_give_beta_c(dtype):
    M, N = 37, 45
    p = inputs.gemm_problem(50, "N", "N", M, N, 8, dtype, "int", scale=4, ld_mode="padded")
    c0 = oracle.decode(p["C"], dtype)
    for K, alpha in ((0, 1.0), (8, 0.0)):
        cbits, _ = run_gemm(p, "N", "N", M, N, K, alpha, 0.5, dtype)
        assert np.array_equal(oracle.decode(cbits[:, :N], dtype), 0.5 * c0[:, :N])
        assert bits_equal(cbits[:, N:], p["C"][:, N:])
    cbits, _ = run_gemm(p, "N", "N", M, N, 0, 1.0, 0.0, dtype)
    assert np.all(oracle.decode(cbits[:, :N], dtype) == 0.0)


def test_beta_one_accumulates_exactly():
    """Integer inputs: gemm(beta=1) on C_old = X equals X + A@B exactly."""
    M, N, K = 130, 200, 96
    p = inputs.gemm_problem(51, "N", "N", M, N, K, "f32", "int", scale=3)
    cbits, _ = run_gemm(p, "N", "N", M, N, K, 1.0, 1.0, "f32")
    ref = oracle.gemm("N", "N", M, N, K, 1.0, p["A"], p["lda"], p["B"], p["ldb"], 1.0, p["C"],
                      p["ldc"], "f32")
    assert np.array_equal(cbits.astype(np.float64), ref)


def test_empty_shapes_are_noops():
    import swiglu_gemm_amd as sg
    C = torch.full((4, 4), 3.0, device="cuda:0")
    A = torch.zeros((4, 4), device="cuda:0")
    for M, N in ((0, 4), (4, 0)):
        sg.gemm(A, A, C, M=M, N=N, K=4, lda=4, ldb=4, ldc=4)
    torch.cuda.synchronize()
    assert torch.all(C == 3.0)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_unaligned_pointers_and_ld(dtype):
    """Operands at odd element offsets with odd leading dimensions take the
    guarded (non-vector) path and must still be correct."""
    import swiglu_gemm_amd as sg
    M, N, K = 150, 133, 77
    gen = np.random.default_rng(21)
    a = inputs.to_storage(gen.standard_normal(1 + M * 79), dtype)
    b = inputs.to_storage(gen.standard_normal(3 + K * 135), dtype)
    c = inputs.to_storage(np.zeros(1 + M * 137), dtype)
    A = to_dev(a, dtype)[1:]
    B = to_dev(b, dtype)[3:]
    C = to_dev(c, dtype)[1:]
    sg.gemm(A, B, C, alpha=1.0, beta=0.0, M=M, N=N, K=K, lda=79, ldb=135, ldc=137,
            dtype={"f16": 1, "bf16": 2}[dtype])
    torch.cuda.synchronize()
    got = oracle.decode(from_dev(C), dtype)[: M * 137].reshape(M, 137)[:, :N]
    Cref = np.zeros(M * 137)
    oracle.gemm_f64("N", "N", M, N, K, 1.0, oracle.decode(a[1:], dtype), 79,
                    oracle.decode(b[3:], dtype), 135, 0.0, Cref, 137)
    assert_close(got, Cref.reshape(M, 137)[:, :N], dtype, K, "unaligned " + sg.last_config())


@pytest.mark.parametrize("tr", ["NN", "TN"])
def test_split_k_skinny(tr):
    """Few output tiles and a long K select split-K; partials are reduced in a
    fixed order before the alpha/beta epilogue."""
    import swiglu_gemm_amd as sg
    M, N, K = 64, 384, 8192
    p = inputs.gemm_problem(52, tr[0], tr[1], M, N, K, "bf16", "normal", ld_mode="padded")
    c1 = check_full(p, tr[0], tr[1], M, N, K, 0.7, 0.3, "bf16", "split-K")
    assert split_count(sg.last_config()) > 1, sg.last_config()
    c2, _ = run_gemm(p, tr[0], tr[1], M, N, K, 0.7, 0.3, "bf16")
    assert bits_equal(c1, c2), "split-K result is not run-to-run identical"


def test_deterministic_large():
    M, N, K = 1024, 1024, 2048
    p = inputs.gemm_problem(53, "N", "N", M, N, K, "f16", "normal", scale=1 / 45.0, beta_zero=True)
    c1, _ = run_gemm(p, "N", "N", M, N, K, 1.0, 0.0, "f16")
    c2, _ = run_gemm(p, "N", "N", M, N, K, 1.0, 0.0, "f16")
    assert bits_equal(c1, c2)


def test_invalid_arguments_do_not_launch():
    import swiglu_gemm_amd as sg
    L = sg.lib()
    import ctypes
    nul = ctypes.c_void_p(0)
    x = torch.zeros(16, device="cuda:0")
    ptr = ctypes.c_void_p(x.data_ptr())
    assert L.sg_gemm(b"X", b"N", 1, 1, 1, 1.0, ptr, 1, ptr, 1, 0.0, ptr, 1, 0, nul) == -1
    assert L.sg_gemm(b"N", b"N", 2, 2, 2, 1.0, ptr, 1, ptr, 2, 0.0, ptr, 2, 0, nul) == -8
    assert L.sg_gemm(b"N", b"N", 2, 2, 2, 1.0, ptr, 2, ptr, 2, 0.0, ptr, 2, 9, nul) == -14
