"""CPU pins of the fp64 oracle against facts the pages and mathematics fix.

Each test checks the oracle against something other than itself: the worked
2x3x2 example printed on "GEMM o Coração Matemático" §1/§2.1, brute force in
exact rational arithmetic, numpy's fp64 matmul (a library routine), algebraic
invariants of §1, closed forms and 50-digit decimal values of SiLU, and torch's
dtype casts for the storage decoders.
"""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from swiglu_gemm_amd import inputs

TRANS = list(itertools.product("NT", "NT"))


def _load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


def _store(X, trans, ld=None):
    """Store op-matrix X (rows x cols) so that op(stored) == X; returns flat, ld."""
    S = X.T if trans == "T" else X
    S = np.ascontiguousarray(S, dtype=np.float64)
    r, c = S.shape
    ld = ld or max(c, 1)
    out = np.full((r, ld), np.nan)
    out[:, :c] = S
    return out.ravel(), ld


# --------------------------------------------------------------------------
# the worked example of §1 / §2.1
# --------------------------------------------------------------------------

def test_worked_example_product_all_orders_and_transposes(golden_dir):
    g = _load(golden_dir, "worked_example_2x3x2.json")
    A = np.array(g["A"], float)
    B = np.array(g["B"], float)
    AB = np.array(g["AB"], float)
    # the printed facts the example is rebuilt from
    assert list(A.ravel()) == g["A_rowmajor_linear"]
    assert A.ravel()[g["A11_linear_position"]] == A[1, 1] == 1
    assert np.array_equal(B.T, np.array(g["B_transpose"], float))
    assert np.array_equal(sum(np.array(o, float) for o in g["outer_products"]), AB)
    for ta, tb in TRANS:
        a, lda = _store(A, ta, ld=5)
        b, ldb = _store(B, tb, ld=4)
        for order in ("ipj", "dot"):
            C = np.full(2 * 3, np.nan)
            oracle.gemm_f64(ta, tb, 2, 2, 3, 1.0, a, lda, b, ldb, 0.0, C, 3, order=order)
            assert np.array_equal(C.reshape(2, 3)[:, :2], AB), (ta, tb, order)
            assert np.isnan(C.reshape(2, 3)[:, 2]).all()   # ld padding untouched


def test_worked_example_alpha_beta(golden_dir):
    g = _load(golden_dir, "worked_example_2x3x2.json")
    A = np.array(g["A"], float).ravel()
    B = np.array(g["B"], float).ravel()
    C = np.array(g["C_old"], float).ravel().copy()
    oracle.gemm_f64("N", "N", 2, 2, 3, g["alpha"], A, 3, B, 2, g["beta"], C, 2)
    assert C[0] == g["C00_printed"] == 17
    assert np.array_equal(C.reshape(2, 2), np.array(g["C_alpha_beta"], float))


def test_worked_example_through_storage_codecs(golden_dir):
    """The same example through every storage dtype's decoder (small integers are
    exact in all of them)."""
    g = _load(golden_dir, "worked_example_2x3x2.json")
    A = np.array(g["A"], float)
    B = np.array(g["B"], float)
    for dt in ("f32", "f16", "bf16", "e4m3"):
        Ab = inputs.to_storage(A, dt)
        Bb = inputs.to_storage(B, dt)
        Cb = inputs.to_storage(np.array(g["C_old"], float), "f32" if dt == "f32" else
                               ("bf16" if dt == "e4m3" else dt))
        cdt = "f32" if dt == "f32" else ("bf16" if dt == "e4m3" else dt)
        C = oracle.gemm("N", "N", 2, 2, 3, 2.0, Ab, 3, Bb, 2, 1.0, Cb, 2, dt, c_dtype=cdt)
        assert np.array_equal(C, np.array(g["C_alpha_beta"], float)), dt


# --------------------------------------------------------------------------
# brute force in exact rational arithmetic
# --------------------------------------------------------------------------

def _fraction_gemm(ta, tb, M, N, K, alpha, As, lda, Bs, ldb, beta, Cs, ldc):
    # build op(A), op(B) explicitly as nested lists, then the textbook sum
    def stored(flat, ld, r, c):
        return [[Fraction(flat[i * ld + j]) for j in range(c)] for i in range(r)]

    if ta == "T":
        S = stored(As, lda, K, M)
        opA = [[S[p][i] for p in range(K)] for i in range(M)]
    else:
        opA = stored(As, lda, M, K)
    if tb == "T":
        S = stored(Bs, ldb, N, K)
        opB = [[S[j][p] for j in range(N)] for p in range(K)]
    else:
        opB = stored(Bs, ldb, K, N)
    out = {}
    for i in range(M):
        for j in range(N):
            s = sum((opA[i][p] * opB[p][j] for p in range(K)), Fraction(0))
            old = Fraction(0) if beta == 0 else Fraction(beta) * Fraction(Cs[i * ldc + j])
            out[i, j] = Fraction(alpha) * s + old
    return out


@pytest.mark.parametrize("ta,tb", TRANS)
def test_bruteforce_fraction_tiny(ta, tb):
    gen = np.random.default_rng(1234)
    for M, N, K in itertools.product((1, 2, 3, 4), (1, 3, 4), (1, 2, 4)):
        ar, ac = (K, M) if ta == "T" else (M, K)
        br, bc = (N, K) if tb == "T" else (K, N)
        lda, ldb, ldc = ac + 1, bc + 2, N + 1
        # dyadic inputs: k/8 with k in [-24, 24]
        As = gen.integers(-24, 25, size=ar * lda) / 8.0
        Bs = gen.integers(-24, 25, size=br * ldb) / 8.0
        Cs = gen.integers(-24, 25, size=M * ldc) / 8.0
        for alpha, beta in ((1.0, 0.0), (0.75, -1.25), (-2.0, 1.0)):
            C = Cs.copy()
            oracle.gemm_f64(ta, tb, M, N, K, alpha, As, lda, Bs, ldb, beta, C, ldc)
            ref = _fraction_gemm(ta, tb, M, N, K, alpha, As, lda, Bs, ldb, beta, Cs, ldc)
            for (i, j), v in ref.items():
                assert Fraction(C[i * ldc + j]) == v, (M, N, K, alpha, beta, i, j)
            for i in range(M):     # padding columns untouched
                assert np.array_equal(C[i * ldc + N:(i + 1) * ldc], Cs[i * ldc + N:(i + 1) * ldc])


# --------------------------------------------------------------------------
# a library routine: numpy fp64 matmul on medium shapes
# --------------------------------------------------------------------------

@pytest.mark.parametrize("ta,tb", TRANS)
def test_against_numpy_matmul(ta, tb):
    gen = np.random.default_rng(7)
    M, N, K = 37, 53, 129
    A = gen.standard_normal((M, K))
    B = gen.standard_normal((K, N))
    C0 = gen.standard_normal((M, N))
    a, lda = _store(A, ta, ld=(M if ta == "T" else K) + 3)
    b, ldb = _store(B, tb, ld=(K if tb == "T" else N) + 5)
    C = np.full((M, N + 2), 7.0)
    C[:, :N] = C0
    C = C.ravel().copy()
    alpha, beta = 0.7, -0.3
    oracle.gemm_f64(ta, tb, M, N, K, alpha, a, lda, b, ldb, beta, C, N + 2)
    ref = alpha * (A @ B) + beta * C0
    got = C.reshape(M, N + 2)[:, :N]
    scale = np.abs(alpha) * (np.abs(A) @ np.abs(B)) + abs(beta) * np.abs(C0)
    assert np.all(np.abs(got - ref) <= 1e-12 * scale)
    assert np.all(C.reshape(M, N + 2)[:, N:] == 7.0)


# --------------------------------------------------------------------------
# algebra of §1
# --------------------------------------------------------------------------

def _int_problem(gen, M, N, K):
    return (gen.integers(-4, 5, size=(M, K)).astype(float),
            gen.integers(-4, 5, size=(K, N)).astype(float))


def test_alpha_commutes_with_product():
    gen = np.random.default_rng(3)
    A, B = _int_problem(gen, 9, 11, 13)
    base = np.zeros(9 * 11)
    oracle.gemm_f64("N", "N", 9, 11, 13, 1.0, A.ravel(), 13, B.ravel(), 11, 0.0, base, 11)
    for alpha in (2.0, 0.5, -4.0, 0.7):
        C = np.zeros(9 * 11)
        oracle.gemm_f64("N", "N", 9, 11, 13, alpha, A.ravel(), 13, B.ravel(), 11, 0.0, C, 11)
        assert np.array_equal(C, alpha * base)   # integer sums: exact for any alpha


def test_beta_zero_ignores_old_c_and_beta_one_accumulates():
    gen = np.random.default_rng(4)
    A, B = _int_problem(gen, 6, 7, 8)
    C = np.full(6 * 7, np.nan)
    oracle.gemm_f64("N", "N", 6, 7, 8, 1.0, A.ravel(), 8, B.ravel(), 7, 0.0, C, 7)
    assert np.isfinite(C).all()
    assert np.array_equal(C.reshape(6, 7), A @ B)
    X = gen.integers(-9, 10, size=(6, 7)).astype(float)
    D = X.ravel().copy()
    oracle.gemm_f64("N", "N", 6, 7, 8, 1.0, A.ravel(), 8, B.ravel(), 7, 1.0, D, 7)
    assert np.array_equal(D.reshape(6, 7), X + C.reshape(6, 7))


def test_alpha_zero_and_k_zero_give_beta_c():
    gen = np.random.default_rng(5)
    X = gen.integers(-9, 10, size=(4, 5)).astype(float)
    A = np.full(4 * 3, np.nan)
    B = np.full(3 * 5, np.nan)
    for K in (0, 3):
        D = X.ravel().copy()
        alpha = 1.0 if K == 0 else 0.0
        if K == 3:
            # alpha == 0 with finite operands (NaN * 0 would be NaN in any reading)
            A = np.ones(4 * 3)
            B = np.ones(3 * 5)
        oracle.gemm_f64("N", "N", 4, 5, K, alpha, A, 3, B, 5, 0.5, D, 5)
        assert np.array_equal(D.reshape(4, 5), 0.5 * X)


def test_identity_and_permutation_are_exact_all_transposes():
    gen = np.random.default_rng(6)
    M, K = 19, 23
    A = gen.standard_normal((M, K))
    perm = gen.permutation(K)
    P = np.zeros((K, K))
    P[np.arange(K), perm] = 1.0       # (A P)[:, perm[p]] = A[:, p]
    for ta, tb in TRANS:
        a, lda = _store(A, ta, ld=(M if ta == "T" else K) + 1)
        for Mat, expect in ((np.eye(K), A), (P, A[:, np.argsort(perm)])):
            b, ldb = _store(Mat, tb, ld=K + 3)
            C = np.zeros(M * K)
            oracle.gemm_f64(ta, tb, M, K, K, 1.0, a, lda, b, ldb, 0.0, C, K)
            assert np.array_equal(C.reshape(M, K), expect), (ta, tb)


def test_op_flag_equals_explicit_transposed_copy():
    gen = np.random.default_rng(8)
    A = gen.standard_normal((10, 12))
    B = gen.standard_normal((12, 9))
    C1 = np.zeros(90)
    C2 = np.zeros(90)
    oracle.gemm_f64("T", "T", 10, 9, 12, 1.0, np.ascontiguousarray(A.T).ravel(), 10,
                    np.ascontiguousarray(B.T).ravel(), 12, 0.0, C1, 9)
    oracle.gemm_f64("N", "N", 10, 9, 12, 1.0, A.ravel(), 12, B.ravel(), 9, 0.0, C2, 9)
    assert np.array_equal(C1, C2)


def test_invalid_arguments_rejected():
    z = np.zeros(4)
    with pytest.raises(ValueError):
        oracle.gemm_f64("X", "N", 1, 1, 1, 1.0, z, 1, z, 1, 0.0, z, 1)
    with pytest.raises(ValueError):
        oracle.gemm_f64("N", "N", -1, 1, 1, 1.0, z, 1, z, 1, 0.0, z, 1)


# --------------------------------------------------------------------------
# SiLU and SwiGLU
# --------------------------------------------------------------------------

def test_silu_closed_forms(golden_dir):
    assert oracle.silu(0.0) == 0.0
    for x in (0.1, 0.5, 1.0, 3.0, 7.25, 15.0):
        # SiLU(x) - SiLU(-x) = x  since sigma(x) + sigma(-x) = 1
        assert abs((oracle.silu(x) - oracle.silu(-x)) - x) <= 4e-16 * x
    assert oracle.silu(50.0) == 50.0                  # -> x as x -> +inf
    assert abs(oracle.silu(-50.0)) < 1e-19            # -> 0 as x -> -inf
    assert oracle.silu(-1000.0) == 0.0                # no overflow to NaN
    g = _load(golden_dir, "silu_decimal.json")
    for v in g["values"]:
        x = float(v["x"])
        ref = float(v["silu"])
        got = oracle.silu(x)
        assert abs(got - ref) <= 4 * np.finfo(float).eps * max(abs(ref), 1e-300), (x, got, ref)


def _interleave_ref(W1, W2):
    K, N = W1.shape
    return np.stack([W1, W2], axis=2).reshape(K, 2 * N)


def test_interleave_layout_and_roundtrip():
    gen = np.random.default_rng(9)
    for dt, K, N in (("bf16", 5, 7), ("e4m3", 3, 4), ("f16", 1, 1), ("f32", 4, 3)):
        W1 = gen.integers(0, 200, size=(K, N)).astype(inputs.STORAGE[dt])
        W2 = gen.integers(0, 200, size=(K, N)).astype(inputs.STORAGE[dt])
        Wf = oracle.interleave(W1, W2)
        assert Wf.shape == (K, 2 * N)
        assert np.array_equal(Wf, _interleave_ref(W1, W2))
        assert np.array_equal(Wf[K - 1, 2 * (N - 1) + 1], W2[K - 1, N - 1])
        assert np.array_equal(Wf[0, 0], W1[0, 0])
        a, b = oracle.deinterleave(Wf)
        assert np.array_equal(a.view(np.uint8), W1.view(np.uint8))
        assert np.array_equal(b.view(np.uint8), W2.view(np.uint8))


def test_swiglu_bruteforce_tiny():
    """Exact rational sums, then SiLU from math.exp: agrees to a few ulps."""
    gen = np.random.default_rng(10)
    M, N, K = 3, 4, 5
    A = gen.integers(-8, 9, size=(M, K)) / 4.0
    W1 = gen.integers(-8, 9, size=(K, N)) / 8.0
    W2 = gen.integers(-8, 9, size=(K, N)) / 8.0
    Wf = _interleave_ref(W1, W2)
    sa, sw = 0.5, 0.25
    Y = oracle.swiglu_f64(M, N, K, A, Wf, sa, sw)
    for m in range(M):
        for n in range(N):
            g = Fraction(sa) * Fraction(sw) * sum(Fraction(A[m, p]) * Fraction(W1[p, n]) for p in range(K))
            u = Fraction(sa) * Fraction(sw) * sum(Fraction(A[m, p]) * Fraction(W2[p, n]) for p in range(K))
            ref = float(g) / (1.0 + math.exp(-float(g))) * float(u)
            assert abs(Y[m, n] - ref) <= 4e-16 * abs(ref) + 1e-300, (m, n)


def test_swiglu_zero_weights_give_zero():
    gen = np.random.default_rng(11)
    M, N, K = 4, 6, 8
    A = gen.standard_normal((M, K))
    W = gen.standard_normal((K, N))
    Z = np.zeros((K, N))
    assert np.all(oracle.swiglu_f64(M, N, K, A, _interleave_ref(Z, W)) == 0.0)
    assert np.all(oracle.swiglu_f64(M, N, K, A, _interleave_ref(W, Z)) == 0.0)


def test_swiglu_one_hot_is_exact_and_detects_swaps():
    """W1, W2 select columns of A (one-hot), so every sum holds one term: Y must be
    exactly SiLU(a_gate) * a_up on the selected entries.  Gate sources are powers
    of two >= 32 (SiLU(g) is g within 2^-46), up sources small integers; swapping
    the gate and up halves changes the result."""
    M, N, K = 5, 6, 16
    gen = np.random.default_rng(12)
    A = np.zeros((M, K))
    A[:, :8] = 2.0 ** gen.integers(5, 9, size=(M, 8))       # gate sources
    A[:, 8:] = gen.integers(-3, 4, size=(M, 8))             # up sources
    pi1 = gen.permutation(8)[:N]
    pi2 = 8 + gen.permutation(8)[:N]
    W1 = np.zeros((K, N))
    W2 = np.zeros((K, N))
    W1[pi1, np.arange(N)] = 1.0
    W2[pi2, np.arange(N)] = 1.0
    Y = oracle.swiglu_f64(M, N, K, A, _interleave_ref(W1, W2))
    g = A[:, pi1]
    u = A[:, pi2]
    assert np.array_equal(Y, g / (1.0 + np.exp(-g)) * u)
    # for g >= 32, SiLU(g) == g to fp64 rounding within 2^-46 relative
    assert np.all(np.abs(Y - g * u) <= 1e-13 * np.abs(g * u))
    # swapping gate/up must change the result
    Ys = oracle.swiglu_f64(M, N, K, A, _interleave_ref(W2, W1))
    assert not np.array_equal(Ys, Y)


def test_swiglu_matches_composition_through_gemm():
    """SwiGLU equals SiLU(GEMM(A,W1)) * GEMM(A,W2), with the GEMMs run through the
    de-interleaved halves; also with a dequantisation scale."""
    gen = np.random.default_rng(13)
    M, N, K = 7, 9, 33
    A = gen.standard_normal((M, K))
    W1 = gen.standard_normal((K, N))
    W2 = gen.standard_normal((K, N))
    Wf = oracle.interleave(W1, W2)
    for sa, sw in ((1.0, 1.0), (0.375, 0.0625)):
        Y = oracle.swiglu_f64(M, N, K, A, Wf, sa, sw)
        G = np.zeros(M * N)
        U = np.zeros(M * N)
        oracle.gemm_f64("N", "N", M, N, K, sa * sw, A.ravel(), K, W1.ravel(), N, 0.0, G, N)
        oracle.gemm_f64("N", "N", M, N, K, sa * sw, A.ravel(), K, W2.ravel(), N, 0.0, U, N)
        ref = G / (1.0 + np.exp(-G)) * U
        assert np.allclose(Y.ravel(), ref, rtol=1e-14, atol=0)
        # and against numpy for the sums
        g = sa * sw * (A @ W1)
        u = sa * sw * (A @ W2)
        assert np.allclose(Y, g / (1 + np.exp(-g)) * u, rtol=1e-12, atol=1e-300)


# --------------------------------------------------------------------------
# storage decoders against torch's casts (a library routine), every code
# --------------------------------------------------------------------------

def _same(a, b):
    return np.array_equal(np.isnan(a), np.isnan(b)) and \
        np.array_equal(a[~np.isnan(a)], b[~np.isnan(b)]) and \
        np.array_equal(np.signbit(a[~np.isnan(a)]), np.signbit(b[~np.isnan(b)]))


def test_decode_every_fp16_code():
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = codes.view(np.float16).astype(np.float64)
    assert _same(oracle.decode(codes, "f16"), ref)


def test_decode_every_bf16_code():
    torch = pytest.importorskip("torch")
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(codes.astype(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert _same(oracle.decode(codes, "bf16"), ref)


def test_decode_every_e4m3_code():
    torch = pytest.importorskip("torch")
    codes = np.arange(256, dtype=np.uint16).astype(np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.decode(codes, "e4m3")
    assert _same(got, ref)
    assert np.nanmax(got) == 448.0 and np.isnan(got).sum() == 2   # S.1111.111


def test_decode_f32_passthrough():
    x = np.array([1.5, -0.0, np.inf, 3.4e38, 1e-45], dtype=np.float32)
    assert _same(oracle.decode(x, "f32"), x.astype(np.float64))
