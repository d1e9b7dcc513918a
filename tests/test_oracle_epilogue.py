"""CPU pins of the oracle's epilogue steps (bias, activation, e4m3 output
quantisation) against facts other than the oracle itself: odd-part identities of
the activations, scipy's erf and the normal CDF (library routines), the 50-digit
SiLU values of tests/golden, the known bound of the tanh form of GELU, numpy's
matmul for the bias/activation wiring, exhaustive code round trips and midpoints
of the e4m3fn grid, and torch's float8_e4m3fn cast."""
import json
import math
import os

import numpy as np
import pytest

import oracle

ACTS = ["relu", "gelu", "gelu_tanh", "silu"]


@pytest.mark.parametrize("act", ACTS)
def test_activation_odd_part_is_identity(act):
    """f(x) - f(-x) = x for x*g(x) with g(x) + g(-x) = 1 (step, Phi, the tanh form,
    the logistic function): catches a wrong sign, a dropped factor 1/2, or erf
    evaluated at x instead of x/sqrt 2."""
    x = np.linspace(-12.0, 12.0, 2401)
    f = oracle.activation(x, act)
    g = oracle.activation(-x, act)
    assert np.allclose(f - g, x, rtol=1e-14, atol=1e-14)


def test_gelu_is_x_times_normal_cdf():
    from scipy.special import erf, erfc
    from scipy.stats import norm
    x = np.linspace(-8.0, 8.0, 1601)
    got = oracle.activation(x, "gelu")
    # full relative accuracy, also in the negative tail where 1 + erf would cancel
    assert np.allclose(got, x * norm.cdf(x), rtol=1e-13, atol=1e-300)
    assert np.allclose(got, 0.5 * x * erfc(-x / np.sqrt(2.0)), rtol=1e-13, atol=1e-300)
    pos = x >= 0
    assert np.allclose(got[pos], 0.5 * x[pos] * (1.0 + erf(x[pos] / np.sqrt(2.0))), rtol=1e-14,
                       atol=1e-300)
    assert oracle.activation(np.array([1.0]), "gelu")[0] == pytest.approx(0.8413447460685429,
                                                                         rel=1e-15)


def test_gelu_tanh_form_stays_within_its_known_bound():
    """The tanh form approximates x*Phi(x) to within a few 1e-4 everywhere."""
    x = np.linspace(-10.0, 10.0, 20001)
    d = np.abs(oracle.activation(x, "gelu_tanh") - oracle.activation(x, "gelu"))
    assert d.max() < 5e-4
    assert d.max() > 1e-5          # it is an approximation, not the same function


def test_silu_matches_the_decimal_golden_values(golden_dir):
    with open(os.path.join(golden_dir, "silu_decimal.json")) as f:
        g = json.load(f)
    pts = g["values"]
    xs = np.array([float(p["x"]) for p in pts])
    want = np.array([float(p["silu"]) for p in pts])
    assert np.allclose(oracle.activation(xs, "silu"), want, rtol=2e-16 * 8, atol=1e-300)


def test_relu_and_none():
    x = np.array([-2.0, -0.0, 0.0, 3.5])
    assert np.array_equal(oracle.activation(x, "relu"), np.array([0.0, 0.0, 0.0, 3.5]))
    assert np.array_equal(oracle.activation(x, "none"), x)


@pytest.mark.parametrize("act", ["none"] + ACTS)
def test_gemm_epilogue_wiring_against_numpy(act):
    """Bias indexed by column (a per-row bias fails: M != N and distinct values),
    added after alpha/beta and before the activation."""
    gen = np.random.default_rng(5)
    M, N, K = 5, 7, 9
    A = gen.standard_normal((M, K)).astype(np.float32)
    B = gen.standard_normal((K, N)).astype(np.float32)
    C = gen.standard_normal((M, N)).astype(np.float32)
    bias = (np.arange(N) - 3.0).astype(np.float32)
    alpha, beta = 0.75, -0.5
    got = oracle.gemm_epilogue("N", "N", M, N, K, alpha, A, K, B, N, beta, C, N, "f32",
                               bias_bits=bias, bias_dtype="f32", act=act)
    pre = alpha * (A.astype(np.float64) @ B.astype(np.float64)) + beta * C + bias[None, :]
    assert np.allclose(got, oracle.activation(pre, act), rtol=1e-12, atol=1e-12)


def test_quantize_roundtrips_every_finite_code():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = oracle.decode(codes, "e4m3")
    for s in (1.0, 0.5, 3.0, 0.013):
        q = oracle.quantize_e4m3(vals * s, s)
        assert np.array_equal(q, codes), s


def test_quantize_midpoints_go_to_the_even_code_and_saturate():
    table = oracle.decode(np.arange(0x7F, dtype=np.uint8), "e4m3")
    mids = (table[:-1] + table[1:]) / 2.0
    q = oracle.quantize_e4m3(mids, 1.0)
    lo = np.arange(0x7E)
    want = np.where(lo % 2 == 0, lo, lo + 1).astype(np.uint8)
    assert np.array_equal(q, want)
    # a hair either side of a midpoint picks the nearer code
    assert np.array_equal(oracle.quantize_e4m3(mids * (1 - 1e-9), 1.0), lo.astype(np.uint8))
    assert np.array_equal(oracle.quantize_e4m3(mids * (1 + 1e-9), 1.0),
                          (lo + 1).astype(np.uint8))
    big = np.array([448.0, 460.0, 464.0, 1e30, np.inf, -500.0, np.nan])
    assert list(oracle.quantize_e4m3(big, 1.0)) == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0x7F]
    assert list(oracle.quantize_e4m3(np.array([0.0, -0.0]), 1.0)) == [0x00, 0x80]


def test_quantize_matches_torch_cast_in_range():
    torch = pytest.importorskip("torch")
    gen = np.random.default_rng(6)
    x = np.concatenate([gen.uniform(-448, 448, 20000), gen.standard_normal(20000) * 0.01,
                        gen.standard_normal(2000) * 1e-3])
    want = torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8)
    got = oracle.quantize_e4m3(x.astype(np.float32).astype(np.float64), 1.0)
    assert np.array_equal(got, want.numpy())
