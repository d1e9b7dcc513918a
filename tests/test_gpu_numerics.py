"""Numerics beside the tolerance gate, through the C ABI against the fp64 oracle.

* Error growth with K against the a-priori bound of a floating-point dot product
  ("GEMM o Coração Matemático" §12.2: with unit roundoff u, a sum of K products in
  floating point is within gamma_K * sum_p |a_p b_p| of the exact sum, gamma_K =
  K u / (1 - K u)).  The library accumulates in fp32 (u = 2^-24) and rounds once to
  the output type (u_out), so every output obeys

      |y - s| <= gamma_{K+1} * S * (1 + u_out) + u_out * |s|,   S = sum_p |a_p b_p|

  (K + 1: fp32 operands' products are rounded too).  The test asserts it with the
  accumulation roundoff doubled (any rounding mode of the partial sums) and records
  how much of the bound the observed error uses.
* The mismatch measure of "Resumo Técnico: Sobreposição de Ativação em Nível de
  Tile ..." (Resultados): the share of outputs more than 1 % off the exact value,
  for the fused kernel and for the unfused path (two GEMMs writing bf16 Gate and Up,
  then SiLU(G) * U), on the bf16 and e4m3 SwiGLU workloads, recorded beside the
  largest errors (the fused kernel's must be the smaller).

With SG_NUMERICS_REPORT=<file> every comparison appends its statistics to that
JSON-lines file."""
import numpy as np
import pytest

import oracle
from swiglu_gemm_amd import inputs
from helpers import assert_close, error_stats, from_dev, record, to_dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

U_ACC = 2.0 ** -24
U_OUT = {"f32": 2.0 ** -24, "f16": 2.0 ** -11, "bf16": 2.0 ** -8}


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import swiglu_gemm_amd as sg
    sg.lib()
    yield


def gamma(k, u):
    return k * u / (1.0 - k * u)


# dtype -> value distribution of the workload that uses it (fp32: U[-1,1]; fp16:
# N(0,1)/sqrt(K); bf16: N(0,1); e4m3: N(0,1) quantised per tensor)
DIST = {"f32": ("uniform", None), "f16": ("normal", "inv_sqrt_k"), "bf16": ("normal", None),
        "e4m3": ("normal", None)}


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16", "e4m3"])
@pytest.mark.parametrize("K", [128, 1024, 8192, 65536])
def test_error_growth_with_k_within_gamma_bound(dtype, K):
    """For e4m3 operands alpha = sA*sB (rounded to fp32) scales the fp32 sum: one more
    fp32 rounding, u*|s|, joins the bound, and the output is bf16."""
    import swiglu_gemm_amd as sg
    M = N = 128
    dist, sc = DIST[dtype]
    scale = 1.0 / np.sqrt(K) if sc == "inv_sqrt_k" else 1.0
    od = "bf16" if dtype == "e4m3" else dtype
    p = inputs.gemm_problem(900 + K, "N", "N", M, N, K, dtype, dist, scale=scale,
                            beta_zero=True, c_dtype=od)
    alpha = oracle.as_f32(p["scale_a"] * p["scale_b"]) if dtype == "e4m3" else 1.0
    A, B, C = to_dev(p["A"], dtype), to_dev(p["B"], dtype), to_dev(p["C"], od)
    print("gamma-bound gemm %s M=%d N=%d K=%d" % (dtype, M, N, K), flush=True)
    sg.gemm(A, B, C, alpha=alpha, beta=0.0,
            dtype={"f32": 0, "f16": 1, "bf16": 2, "e4m3": 3}[dtype])
    torch.cuda.synchronize()
    desc = sg.last_config()
    y = oracle.decode(from_dev(C), od)
    a = oracle.decode(p["A"], dtype)
    b = oracle.decode(p["B"], dtype)
    s = np.zeros((M, N))
    oracle.gemm_f64("N", "N", M, N, K, alpha, a.ravel(), p["lda"], b.ravel(), p["ldb"], 0.0,
                    s.ravel(), N)
    S = np.zeros((M, N))
    oracle.gemm_f64("N", "N", M, N, K, alpha, np.abs(a).ravel(), p["lda"], np.abs(b).ravel(),
                    p["ldb"], 0.0, S.ravel(), N)
    err = np.abs(y - s)
    uo = U_OUT[od]
    ua = U_ACC if dtype == "e4m3" else 0.0          # the fp32 product alpha * sum
    bound = gamma(K + 1, U_ACC) * S * (1 + uo) * (1 + ua) + (uo + ua) * np.abs(s)
    bound2 = gamma(K + 1, 2 * U_ACC) * S * (1 + uo) * (1 + ua) + (uo + ua) * np.abs(s)
    assert np.all(np.isfinite(y)), desc
    worst = float(np.max(err / bound2))
    assert worst <= 1.0, "%s K=%d %s: error %.3g of the bound" % (dtype, K, desc, worst)
    st = error_stats(y, s, od, K)
    st.update(config=desc, rms_abs=float(np.sqrt(np.mean(err ** 2))),
              err_over_gamma_bound=float(np.max(err / bound)),
              err_over_gamma_k_S=float(np.max(err / (gamma(K, U_ACC) * S))),
              gamma_k=gamma(K, U_ACC))
    record("gamma-bound %s K=%d" % (dtype, K), st)


def unfused_swiglu(A, W1, W2, M, N, dtype, alpha):
    """Two GEMMs writing bf16 Gate and Up to memory, then SiLU(G) * U: the unfused
    composition the fused kernel replaces."""
    import swiglu_gemm_amd as sg
    G = torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0")
    U = torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0")
    Y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0")
    code = {"bf16": 2, "e4m3": 3}[dtype]
    sg.gemm(A, W1, G, alpha=alpha, dtype=code)
    sg.gemm(A, W2, U, alpha=alpha, dtype=code)
    sg.silu_mul(G, U, Y)
    return Y


@pytest.mark.parametrize("dtype,M", [("bf16", 128), ("bf16", 512), ("bf16", 2048),
                                     ("e4m3", 1), ("e4m3", 16), ("e4m3", 256)])
def test_mismatch_share_fused_vs_unfused(dtype, M):
    import swiglu_gemm_amd as sg
    N, K = (4864, 896) if dtype == "bf16" else (11008, 4096)
    pb = inputs.swiglu_problem(4 if dtype == "bf16" else 5, M, N, K, dtype)
    sa, sw = pb["scale_a"], pb["scale_w"]
    Wf = oracle.interleave(pb["W1"], pb["W2"])
    A = to_dev(pb["A"], dtype)
    Y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda:0")
    print("mismatch swiglu %s M=%d" % (dtype, M), flush=True)
    sg.swiglu_gemm(A, to_dev(Wf, dtype), Y, sa, sw)
    fused_desc = sg.last_config()
    Yu = unfused_swiglu(A, to_dev(pb["W1"], dtype), to_dev(pb["W2"], dtype), M, N, dtype,
                        sa * sw)
    torch.cuda.synchronize()
    ref = oracle.swiglu(M, N, K, pb["A"], Wf, dtype, sa, sw)
    yf = oracle.decode(from_dev(Y), "bf16")
    yu = oracle.decode(from_dev(Yu), "bf16")
    assert_close(yf, ref, dtype, K, "fused " + fused_desc)
    sf = error_stats(yf, ref, dtype, K)
    su = error_stats(yu, ref, dtype, K)
    record("swiglu %s M=%d fused" % (dtype, M), dict(sf, config=fused_desc))
    record("swiglu %s M=%d unfused" % (dtype, M), su)
    # one rounding of the fp32 result against three (Gate, Up, then the product): the
    # largest error of the fused kernel is the smaller one.  The >1 % shares are
    # recorded only: they count outputs near zero, where any rounding is a large
    # relative error.
    assert sf["max_abs"] <= su["max_abs"], (sf, su)
