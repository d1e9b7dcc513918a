"""sg_gemm_noalloc through the C ABI: the entry point for callers that cannot
allocate device memory gives the same bits as sg_gemm on problems whose kernels
use scratch memory (split-K partial sums; the decode path's partial sums; e4m3
operands re-laid with 16-byte rows), on two calls in a row with the second one
smaller, and refuses a problem that needs more than its fixed scratch before
enqueuing anything."""
import ctypes
import os

import numpy as np
import pytest

import oracle
from swiglu_gemm_amd import inputs
from helpers import assert_close, bits_equal, from_dev, split_count, to_dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

SCRATCH_LIMIT = -100                     # SG_STATUS_SCRATCH_LIMIT
SCRATCH_BYTES = 32 << 20                 # SG_NOALLOC_SCRATCH_BYTES


@pytest.fixture(scope="module")
def L():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import swiglu_gemm_amd as sg
    yield sg.lib()
    os.environ.pop("SG_FORCE_CONFIG", None)


def call(L, fn, p, ta, tb, M, N, K, alpha, beta, dtype, C):
    import swiglu_gemm_amd as sg
    code = {"f16": 1, "bf16": 2, "e4m3": 3}[dtype]
    A, B = to_dev(p["A"], dtype), to_dev(p["B"], dtype)
    st = getattr(L, fn)(ta.encode(), tb.encode(), M, N, K, alpha, ctypes.c_void_p(A.data_ptr()),
                        p["lda"], ctypes.c_void_p(B.data_ptr()), p["ldb"], beta,
                        ctypes.c_void_p(C.data_ptr()), p["ldc"], code,
                        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    return st, sg.last_config()


def same_as_sg_gemm(L, ta, tb, M, N, K, dtype, seed, beta=0.0):
    """sg_gemm_noalloc and sg_gemm on one problem: identical bits, within tolerance of
    the oracle; returns the configuration description."""
    p = inputs.gemm_problem(seed, ta, tb, M, N, K, dtype, "normal", ld_mode="padded",
                            beta_zero=beta == 0.0)
    print("noalloc %s %s%s M=%d N=%d K=%d" % (dtype, ta, tb, M, N, K), flush=True)
    C1 = to_dev(p["C"], dtype)
    st, desc = call(L, "sg_gemm_noalloc", p, ta, tb, M, N, K, 0.7, beta, dtype, C1)
    assert st == 0, (st, desc)
    C2 = to_dev(p["C"], dtype)
    st2, desc2 = call(L, "sg_gemm", p, ta, tb, M, N, K, 0.7, beta, dtype, C2)
    assert st2 == 0 and desc2 == desc, (desc, desc2)
    c1 = from_dev(C1)
    assert bits_equal(c1, from_dev(C2)), desc
    ref = oracle.gemm(ta, tb, M, N, K, 0.7, p["A"], p["lda"], p["B"], p["ldb"], beta, p["C"],
                      p["ldc"], dtype)
    assert_close(oracle.decode(c1, dtype)[:, :N], ref[:, :N], dtype, K, desc)
    assert bits_equal(c1[:, N:], p["C"][:, N:]), "ld padding written"
    return desc


def test_split_k_twice_second_smaller(L):
    d1 = same_as_sg_gemm(L, "N", "T", 96, 4096, 4096, "bf16", 700, beta=0.25)
    assert split_count(d1) > 1, d1
    d2 = same_as_sg_gemm(L, "N", "T", 64, 4096, 4096, "bf16", 701)
    assert split_count(d2) > 1, d2


def test_decode_path_twice_second_smaller(L):
    d1 = same_as_sg_gemm(L, "N", "N", 8, 4096, 4096, "f16", 702)
    assert "decode" in d1 and "fixup" in d1, d1
    d2 = same_as_sg_gemm(L, "N", "T", 3, 2048, 4096, "bf16", 703)
    assert "decode" in d2 and "fixup" in d2, d2


def test_too_large_is_refused_before_any_launch(L):
    """16 splits of a 1024 x 4096 fp32 partial tile need 256 MiB: refused, C intact."""
    M, N, K = 1024, 4096, 8192
    p = inputs.gemm_problem(704, "N", "N", M, N, K, "bf16", "normal", beta_zero=False)
    assert 16 * M * N * 4 > SCRATCH_BYTES
    C = to_dev(p["C"], "bf16")
    os.environ["SG_FORCE_CONFIG"] = "13,16"
    try:
        st, _ = call(L, "sg_gemm_noalloc", p, "N", "N", M, N, K, 1.0, 0.5, "bf16", C)
    finally:
        os.environ.pop("SG_FORCE_CONFIG", None)
    assert st == SCRATCH_LIMIT, st
    assert bits_equal(from_dev(C), p["C"])
    import swiglu_gemm_amd as sg
    assert "scratch" in sg.status_string(st)
    # in its default configuration the same problem fits, and matches sg_gemm
    st2, desc = call(L, "sg_gemm_noalloc", p, "N", "N", M, N, K, 1.0, 0.5, "bf16", C)
    assert st2 == 0, (st2, desc)
    C2 = to_dev(p["C"], "bf16")
    st3, desc3 = call(L, "sg_gemm", p, "N", "N", M, N, K, 1.0, 0.5, "bf16", C2)
    assert st3 == 0 and desc3 == desc and bits_equal(from_dev(C), from_dev(C2)), desc


def e4m3_both(L, M, N, K, seed):
    """One e4m3 problem with tight leading dimensions (rows off the 16-byte grid)
    through sg_gemm_noalloc and sg_gemm; each output within tolerance of the oracle.
    Returns both descriptions and outputs."""
    p = inputs.gemm_problem(seed, "N", "N", M, N, K, "e4m3", "normal", ld_mode="tight",
                            beta_zero=True, c_dtype="bf16")
    alpha = p["scale_a"] * p["scale_b"]
    ref = oracle.gemm("N", "N", M, N, K, alpha, p["A"], p["lda"], p["B"], p["ldb"], 0.0, p["C"],
                      p["ldc"], "e4m3", c_dtype="bf16")
    out = []
    for fn in ("sg_gemm_noalloc", "sg_gemm"):
        print("%s e4m3 M=%d N=%d K=%d" % (fn, M, N, K), flush=True)
        C = to_dev(p["C"], "bf16")
        st, desc = call(L, fn, p, "N", "N", M, N, K, alpha, 0.0, "e4m3", C)
        assert st == 0, (fn, st, desc)
        c = from_dev(C)
        assert_close(oracle.decode(c, "bf16"), ref, "e4m3", K, "%s %s" % (fn, desc))
        out.append((desc, c))
    return out


def test_e4m3_relaid_operands_twice_second_smaller(L):
    """e4m3 rows off the 16-byte grid are re-laid in the fixed scratch next to the
    split-K partial sums (two pieces of it in one call): same bits as sg_gemm."""
    (d1, c1), (d2, c2) = e4m3_both(L, 40, 300, 4100, 705)
    assert d1 == d2 and "gemm8 cfg=" in d1 and split_count(d1) > 1, (d1, d2)
    assert bits_equal(c1, c2), d1
    (d1, c1), (d2, c2) = e4m3_both(L, 37, 80, 70, 706)
    assert d1 == d2 and "gemm8 cfg=" in d1, (d1, d2)
    assert bits_equal(c1, c2), d1


def test_e4m3_relay_beyond_scratch_takes_generic_kernel(L):
    """A 4100 x 8200 e4m3 A with rows off the 16-byte grid needs a 33.7 MB copy,
    more than the fixed scratch: sg_gemm_noalloc runs the generic kernel instead
    (no failure), sg_gemm the tile kernels; both within tolerance of the oracle."""
    assert 4100 * 8208 > SCRATCH_BYTES
    (d1, _), (d2, _) = e4m3_both(L, 4100, 8, 8200, 707)
    assert "generic" in d1, d1
    assert "gemm8 cfg=" in d2, d2


def test_argument_checks_match_sg_gemm(L):
    P = ctypes.c_void_p(16)
    for fn in ("sg_gemm", "sg_gemm_noalloc"):
        f = getattr(L, fn)
        assert f(b"X", b"N", 4, 4, 4, 1.0, P, 4, P, 4, 0.0, P, 4, 1, None) == -1
        assert f(b"N", b"N", 4, 4, 4, 1.0, P, 4, P, 4, 0.0, P, 3, 1, None) == -13
        assert f(b"N", b"N", 0, 4, 4, 1.0, P, 4, P, 4, 0.0, P, 4, 1, None) == 0
